// Exact comparison of two dot-product ratios in integer arithmetic, for the
// decision float64 cannot certify in the SimHash probe order: which of two
// hyperplanes is nearer to x, |x.a| / |a| against |x.b| / |b|.
//
// Every stored value is m 2^e with an integer significand m (bf16: |m| < 2^8;
// float32: |m| < 2^24), so a dot product or a squared norm is an integer
// times a power of two.  They are accumulated into little-endian 32-bit limbs
// at a chosen base exponent, squared and multiplied, all in a caller-given
// word array (LDS); one lane does the work.  A comparison whose integers need
// more words than the array holds returns kExactNoRoom.
#pragma once

#include "common.h"

namespace fastar {

constexpr int kExactNoRoom = 2;

template <typename T> struct ExactVal;
template <> struct ExactVal<uint16_t> {  // bf16 bits
  static constexpr int kSigBits = 8;
  static __device__ __forceinline__ void split(uint16_t h, int64_t& m, int& e) {
    const int ex = (h >> 7) & 0xFF, fr = h & 0x7F;
    m = ex ? (fr | 0x80) : fr;
    e = (ex ? ex : 1) - 134;  // (1 + fr / 2^7) 2^(ex - 127), or fr 2^-133
    if (h & 0x8000) m = -m;
  }
};
template <> struct ExactVal<float> {
  static constexpr int kSigBits = 24;
  static __device__ __forceinline__ void split(float f, int64_t& m, int& e) {
    const uint32_t u = __float_as_uint(f);
    const int ex = (u >> 23) & 0xFF;
    const int64_t fr = u & 0x7FFFFF;
    m = ex ? (fr | 0x800000) : fr;
    e = (ex ? ex : 1) - 150;  // (1 + fr / 2^23) 2^(ex - 127), or fr 2^-149
    if (u >> 31) m = -m;
  }
};

// v[0 .. n) += val 2^bit (the sum fits in n limbs)
__device__ inline void big_add_shifted(uint32_t* v, int n, uint64_t val, int bit) {
  int k = bit >> 5;
  const int sh = bit & 31;
  const uint64_t lo = val << sh;
  const uint32_t w[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), sh ? (uint32_t)(val >> (64 - sh)) : 0u};
  uint64_t carry = 0;
  #pragma unroll 1
  for (int i = 0; k < n && (i < 3 || carry); ++i, ++k) {
    const uint64_t t = (uint64_t)v[k] + (i < 3 ? w[i] : 0u) + carry;
    v[k] = (uint32_t)t;
    carry = t >> 32;
  }
}
// -1, 0, 1 as a < b, a == b, a > b (n limbs each)
__device__ inline int big_cmp(const uint32_t* a, const uint32_t* b, int n) {
  #pragma unroll 1
  for (int i = n - 1; i >= 0; --i)
    if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
  return 0;
}
// a -= b (a >= b)
__device__ inline void big_sub(uint32_t* a, const uint32_t* b, int n) {
  int64_t borrow = 0;
  #pragma unroll 1
  for (int i = 0; i < n; ++i) {
    const int64_t t = (int64_t)a[i] - b[i] - borrow;
    a[i] = (uint32_t)t;
    borrow = t < 0 ? 1 : 0;
  }
}
__device__ inline bool big_zero(const uint32_t* a, int n) {
  #pragma unroll 1
  for (int i = 0; i < n; ++i)
    if (a[i]) return false;
  return true;
}
// c[0 .. na + nb) = a[0 .. na) b[0 .. nb)
__device__ inline void big_mul(uint32_t* c, const uint32_t* a, int na, const uint32_t* b, int nb) {
  #pragma unroll 1
  for (int i = 0; i < na + nb; ++i) c[i] = 0u;
  #pragma unroll 1
  for (int i = 0; i < na; ++i) {
    uint64_t carry = 0;
    #pragma unroll 1
    for (int j = 0; j < nb; ++j) {
      const uint64_t t = (uint64_t)a[i] * b[j] + c[i + j] + carry;
      c[i + j] = (uint32_t)t;
      carry = t >> 32;
    }
    c[i + nb] = (uint32_t)carry;
  }
}
// limbs for integers whose terms span exponents [e0, e1] with 2 kSigBits-bit
// significands, up to 2^8 terms, at base e0
template <typename T>
__device__ __forceinline__ int big_limbs(int e0, int e1) {
  return (e1 - e0 + 2 * ExactVal<T>::kSigBits + 8 + 31) / 32 + 1;
}

// |x . y| into s (n limbs, base e0; tmp: n words of scratch); returns the
// sign of x . y
template <typename T, int D>
__device__ int big_dot(const T* x, const T* y, uint32_t* s, uint32_t* tmp, int n, int e0) {
  using EV = ExactVal<T>;
  #pragma unroll 1
  for (int i = 0; i < n; ++i) s[i] = tmp[i] = 0u;
  #pragma unroll 1
  for (int d = 0; d < D; ++d) {
    int64_t mx, my;
    int ex, ey;
    EV::split(x[d], mx, ex);
    EV::split(y[d], my, ey);
    if (!mx || !my) continue;
    const int64_t pr = mx * my;  // |pr| < 2^(2 kSigBits)
    big_add_shifted(pr > 0 ? s : tmp, n, (uint64_t)(pr > 0 ? pr : -pr), ex + ey - e0);
  }
  const int c = big_cmp(s, tmp, n);
  if (c >= 0) {
    big_sub(s, tmp, n);
  } else {
    big_sub(tmp, s, n);
    #pragma unroll 1
    for (int i = 0; i < n; ++i) s[i] = tmp[i];
  }
  return c;
}
// |x|^2 into q (m limbs, base f0)
template <typename T, int D>
__device__ void big_sqnorm(const T* x, uint32_t* q, int m, int f0) {
  using EV = ExactVal<T>;
  #pragma unroll 1
  for (int i = 0; i < m; ++i) q[i] = 0u;
  #pragma unroll 1
  for (int d = 0; d < D; ++d) {
    int64_t mx;
    int ex;
    EV::split(x[d], mx, ex);
    if (mx) big_add_shifted(q, m, (uint64_t)(mx * mx), 2 * ex - f0);
  }
}
// exponent range of the nonzero products x_i y_i (lo = INT_MAX: none)
template <typename T, int D>
__device__ void prod_exp_range(const T* x, const T* y, int& lo, int& hi) {
  using EV = ExactVal<T>;
  #pragma unroll 1
  for (int d = 0; d < D; ++d) {
    int64_t mx, my;
    int ex, ey;
    EV::split(x[d], mx, ex);
    EV::split(y[d], my, ey);
    if (mx && my) lo = min(lo, ex + ey), hi = max(hi, ex + ey);
  }
}

// For one vector x and two vectors a, b: the sign of
// (x.a)^2 |b|^2 - (x.b)^2 |a|^2, and (if sa, sb are given) the signs of x.a
// and x.b.  Returns kExactNoRoom when cap words are too few (9 n + 4 m, for
// n-limb dot products and m-limb squared norms) or a or b is zero (then
// *sa / *sb are not set).
template <typename T, int D>
__device__ int exact_ratio_cmp(const T* x, const T* a, const T* b, uint32_t* W, int cap, int* sa, int* sb) {
  int e0 = INT_MAX, e1 = INT_MIN, f0 = INT_MAX, f1 = INT_MIN;
  prod_exp_range<T, D>(x, a, e0, e1);
  prod_exp_range<T, D>(x, b, e0, e1);
  prod_exp_range<T, D>(a, a, f0, f1);
  prod_exp_range<T, D>(b, b, f0, f1);
  if (f0 == INT_MAX) return kExactNoRoom;  // both zero
  if (e0 == INT_MAX) {                      // both dot products exactly 0
    if (sa) *sa = 0;
    if (sb) *sb = 0;
    return 0;
  }
  const int n = big_limbs<T>(e0, e1), m = big_limbs<T>(f0, f1);
  if (9 * n + 4 * m > cap) return kExactNoRoom;
  uint32_t* da = W;            // |x.a|   n
  uint32_t* db = da + n;       // |x.b|   n
  uint32_t* tn = db + n;       // scratch n
  uint32_t* na = tn + n;       // |a|^2   m
  uint32_t* nb = na + m;       // |b|^2   m
  uint32_t* sq = nb + m;       // a square   2n
  uint32_t* pa = sq + 2 * n;   // (x.a)^2 |b|^2   2n + m
  uint32_t* pb = pa + 2 * n + m;
  const int ga = big_dot<T, D>(x, a, da, tn, n, e0);
  const int gb = big_dot<T, D>(x, b, db, tn, n, e0);
  big_sqnorm<T, D>(a, na, m, f0);
  big_sqnorm<T, D>(b, nb, m, f0);
  if (big_zero(na, m) || big_zero(nb, m)) return kExactNoRoom;
  if (sa) *sa = ga;
  if (sb) *sb = gb;
  big_mul(sq, da, n, da, n);
  big_mul(pa, sq, 2 * n, nb, m);
  big_mul(sq, db, n, db, n);
  big_mul(pb, sq, 2 * n, na, m);
  return big_cmp(pa, pb, 2 * n + m);
}

}  // namespace fastar
