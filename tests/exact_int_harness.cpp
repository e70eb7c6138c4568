// Host build of the exact ratio comparison (csrc/exact_int.h) for the CPU
// tests: the header is included with its device qualifiers defined away.
// Input: records of {dtype (0 bf16 bits, 1 float32), dim, cap} followed by
// the vectors x, a, b; output: one result per record.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>
using std::max;
using std::min;
#define __device__
#define __forceinline__ inline
static inline uint32_t __float_as_uint(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
#include "exact_int_host.h"

template <typename T, int D>
static bool run(FILE* f, int cap) {
  std::vector<T> x(D), a(D), b(D);
  if (fread(x.data(), sizeof(T), D, f) != (size_t)D || fread(a.data(), sizeof(T), D, f) != (size_t)D ||
      fread(b.data(), sizeof(T), D, f) != (size_t)D)
    return false;
  std::vector<uint32_t> W(cap > 0 ? cap : 1);
  printf("%d\n", fastar::exact_ratio_cmp<T, D>(x.data(), a.data(), b.data(), W.data(), cap, nullptr, nullptr));
  return true;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int hdr[3];
  while (fread(hdr, 4, 3, f) == 3) {
    const int dt = hdr[0], D = hdr[1], cap = hdr[2];
    bool ok;
    if (dt == 0) ok = D == 128 ? run<uint16_t, 128>(f, cap) : run<uint16_t, 64>(f, cap);
    else ok = D == 128 ? run<float, 128>(f, cap) : run<float, 64>(f, cap);
    if (!ok) return 3;
  }
  fclose(f);
  return 0;
}
