// Shared device helpers for the libfastar kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastar.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

#define FASTAR_WAVE 64

// s_waitcnt immediate: vector memory count 0, the other counters unconstrained
constexpr int kWaitVm0 = 0x0F70;

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// launch order.  xcd_block maps launch index i of a 1-D grid of
// 8 * xcd_span(n) workgroups to logical block i % 8 * xcd_span(n) + i / 8, so
// that each XCD runs one contiguous range of logical blocks and neighbouring
// blocks, which tend to read the same rows, share an L2.  Logical blocks >= n
// are empty.
#define FASTAR_XCDS 8

// probes per LSH table (FASTAR_MAX_PROBES)
constexpr int kMaxProbes = FASTAR_MAX_PROBES;
__host__ __device__ __forceinline__ int64_t xcd_span(int64_t n) {
  return (n + FASTAR_XCDS - 1) / FASTAR_XCDS;
}
__device__ __forceinline__ int64_t xcd_block(int64_t i, int64_t n) {
  return (i % FASTAR_XCDS) * xcd_span(n) + i / FASTAR_XCDS;
}

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// round-to-nearest-even float32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two float32 rounded to nearest-even bf16 by one v_cvt_pk_bf16_f32; lo in
// bits 0..15 (finite inputs: the same bits as f32_to_bf16_bits)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) {
    p[i] = (uint16_t)f32_to_bf16_bits(v);
  }
};

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (FASTAR_WAVE - 1); }

// A workgroup barrier that orders LDS accesses only: global loads and stores
// still in flight stay in flight (__syncthreads waits for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, FASTAR_WAVE); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, FASTAR_WAVE); }

// v combined with v of lane ^ 16 (lane ^ 32) without LDS: a permlane swap
// hands every lane both values, in an order that depends on the lane, so
// only commutative combines are offered
__device__ __forceinline__ f32x2_t pair_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (f32x2_t){__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2_t pair_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return (f32x2_t){__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// the value of lane l ^ 16 (either word of the swap may be this lane's own
// value; where both words are equal, they are the partner's as well)
__device__ __forceinline__ uint32_t xor16_word(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] == v ? r[1] : r[0];
}
__device__ __forceinline__ float max_xor16(float v) { const f32x2_t p = pair_xor16(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max_xor32(float v) { const f32x2_t p = pair_xor32(v); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor16(float v) { const f32x2_t p = pair_xor16(v); return p.x + p.y; }
__device__ __forceinline__ float sum_xor32(float v) { const f32x2_t p = pair_xor32(v); return p.x + p.y; }
__device__ __forceinline__ uint32_t or_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] | r[1];
}
__device__ __forceinline__ uint32_t or_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] | r[1];
}

// a commutative, associative combine over the wave without LDS: DPP pairs
// within quads (lane ^ 1, lane ^ 2), then each half-row and row with its
// mirror image, then the permlane swaps across rows
template <typename Op>
__device__ __forceinline__ int wave_reduce_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = op((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return op((int)r[0], (int)r[1]);
}
// inclusive prefix sum over the wave without LDS: shifts within rows of 16
// (lanes shifted in from outside the row add 0), then each row adds the
// totals of the rows before it (row_bcast:15 to rows 1 and 3, row_bcast:31
// to rows 2 and 3)
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}
__device__ __forceinline__ int wave_min_dpp(int v) {
  return wave_reduce_dpp(v, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_sum_dpp(int v) {
  return wave_reduce_dpp(v, [](int a, int b) { return a + b; });
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------
// error-free transformations for exact sign evaluation (Knuth TwoSum; Shewchuk,
// "Adaptive precision floating-point arithmetic and fast robust geometric
// predicates", 1997: Grow-Expansion with zero elimination).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bv = s - a;
  double av = s - bv;
  e = (a - av) + (b - bv);
}

// Adds b to the nonoverlapping expansion e[0..m) (increasing magnitude);
// returns the new length.  e must have room for m + 1 components.
__device__ inline int grow_expansion(double* e, int m, double b) {
  double q = b;
  int k = 0;
  for (int i = 0; i < m; ++i) {
    double s, h;
    two_sum(q, e[i], s, h);
    q = s;
    if (h != 0.0) e[k++] = h;
  }
  if (q != 0.0 || k == 0) e[k++] = q;
  return k;
}

// sign of an expansion: the sign of its largest nonzero component
__device__ inline int expansion_sign(const double* e, int m) {
  for (int i = m - 1; i >= 0; --i) {
    if (e[i] > 0.0) return 1;
    if (e[i] < 0.0) return -1;
  }
  return 0;
}
