// Shared device helpers for the libfastar kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastar.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

#define FASTAR_WAVE 64

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// launch order.  xcd_block maps launch index i of a 1-D grid of
// 8 * xcd_span(n) workgroups to logical block i % 8 * xcd_span(n) + i / 8, so
// that each XCD runs one contiguous range of logical blocks and neighbouring
// blocks, which tend to read the same rows, share an L2.  Logical blocks >= n
// are empty.
#define FASTAR_XCDS 8
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

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, FASTAR_WAVE); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, FASTAR_WAVE); }

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
