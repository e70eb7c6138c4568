// TempCache with quantized ANN matching on gfx950 (paperlayer.ai section 5
// "ANN Attention": LSH or quantized similarity search, no offline
// preprocessing; appendix C, quantization precision; paper.rainbus.top,
// reproducibility: 8-bit by default).
//
// Every key is coded on its own row scale, symmetric, to b-bit integers:
// c_i = round_half_even(Q x_i / max_i |x_i|), Q = 2^(b-1) - 1; the cosine of
// the decoded rows equals the cosine of the integer codes.  A new key of
// frame f is matched against every token of frame f - 1 (for f = 0 the
// frontier's representatives): its best candidate by code cosine (ties to the
// smaller index), proposed if that cosine passes tau; each candidate keeps
// its best proposer (ties to the smaller key).  Launches:
//   tcq_encode   the codes of table 0 (the frontier) and tables 1..F (the new
//                frames), their squared norms, 1 / norms and candidate biases
//                (-inf: no candidate); clears the successor links and the
//                opener counts;
//   tcq_match    per (frame, head, 64 keys): the code dot products of every
//                key with every candidate on int8 MFMA
//                (v_mfma_i32_16x16x64_i8), a running float32 top-2 per key;
//                a decision the float32 bound cannot certify is redone
//                exactly in integers by the whole wave;
//   tcq_resolve  per (frame, head): the proposals grouped by candidate, the
//                best proposer wins (float32 screening, exact compares), links,
//                successor links and opener counts;
//   then the same group updates and representatives' index as the LSH match.
//
// Exact codes.  bf16 x: Q x is exact in float32 (8 + 7 significant bits) and
// the quotient by m = max |x| is correctly rounded (__fdiv_rn).  Writing
// x = a 2^e, m = b 2^g with 8-bit integer significands, a quotient that is not
// a half-integer k + 1/2 differs from it by at least 2^(e-g) / (2 b), which is
// at least 2^23 / (Q a) >= 259 half-ulps of the quotient: its rounding cannot
// cross k + 1/2, and an exact half-integer is representable, so rintf (ties to
// even) gives the exact rounding.  float32 x: the same argument in float64
// (Q x exact in 31 bits; at least 2^52 / (Q a) half-ulps).

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

typedef int v4i32_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// codes
// ---------------------------------------------------------------------------
struct EncArgs {
  // mode 0: the rows of x [H][N][D]; mode 1: the merge's tables 0..F
  int mode, H, bits;
  const void* x;
  int64_t sh, st, N;
  // mode 1
  const void* rep_k;        // [H][cap][D] (table 0 rows through the frontier)
  const int32_t* frontier;  // [H][T]
  const int32_t* n_groups;  // [H]
  int T, F, cap;
  int32_t* nextj;           // [H][F][T], cleared to -1
  int32_t* ocnt;            // [H][nblk + 1], cleared; [nblk] = n_groups
  int nblk;
  // query-driven: tables F + 1 .. 2F are the new frames' queries
  const void* q;
  int64_t qsh, qst;
  int qd;
  // outputs
  int8_t* codes;
  int32_t* norm2;
  float* rn;
  float* bias;
};

template <typename T>
__device__ __forceinline__ int quant_elem(float x, float m, int q);
template <>
__device__ __forceinline__ int quant_elem<uint16_t>(float x, float m, int q) {
  return (int)__builtin_rintf(__fdiv_rn((float)q * x, m));
}
template <>
__device__ __forceinline__ int quant_elem<float>(float x, float m, int q) {
  return (int)__builtin_rint(((double)q * (double)x) / (double)m);
}

// 16 lanes per row (D / 16 elements each), 16 rows per workgroup; grid (row
// blocks, tables, heads) (mode 0: one table of N rows), so that no thread
// divides to find its row; the threads also clear the successor links and
// opener counts (mode 1)
template <typename T, int D>
__global__ __launch_bounds__(256) void tcq_encode_kernel(EncArgs e) {
  constexpr int EPL = D / 16;
  const int sub = threadIdx.x & 15;
  const int ntab = e.F + 1 + (e.qd ? e.F : 0);
  const int h = blockIdx.z, t = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // the row within its table
  if (e.mode == 1) {
    const int64_t blk = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t gid = blk * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
    for (int64_t j = gid; j < (int64_t)e.H * e.F * e.T; j += stride) e.nextj[j] = -1;
    const int nob = e.H * (e.nblk + 1);
    for (int64_t j = gid; j < nob; j += stride) {
      const int hh = (int)j / (e.nblk + 1);
      const int b = (int)j - hh * (e.nblk + 1);
      e.ocnt[j] = b < e.nblk ? 0 : e.n_groups[hh];
    }
  }
  if (i >= (e.mode == 0 ? e.N : (int64_t)e.T)) return;  // 16 whole lanes of a row
  // the row's index in the code table [H][tables][rows]
  const int64_t r = e.mode == 0 ? (int64_t)h * e.N + i : ((int64_t)h * ntab + t) * e.T + i;
  const T* src = nullptr;
  bool valid = true;
  if (e.mode == 0) {
    src = (const T*)e.x + (int64_t)h * e.sh + i * e.st;
  } else {
    if (t == 0) {
      const int g = e.frontier[(int64_t)h * e.T + i];
      valid = e.n_groups[h] > 0 && g >= 0 && g < e.cap;
      src = (const T*)e.rep_k + ((int64_t)h * e.cap + (valid ? g : 0)) * D;
    } else if (t <= e.F) {
      src = (const T*)e.x + (int64_t)h * e.sh + ((int64_t)(t - 1) * e.T + i) * e.st;
    } else {
      src = (const T*)e.q + (int64_t)h * e.qsh + ((int64_t)(t - 1 - e.F) * e.T + i) * e.qst;
    }
  }
  float v[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) v[k] = valid ? Elem<T>::load(src, sub * EPL + k) : 0.f;
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) m = fmaxf(m, fabsf(v[k]));
  m = fmaxf(m, shfl_xor_f(m, 1));
  m = fmaxf(m, shfl_xor_f(m, 2));
  m = fmaxf(m, shfl_xor_f(m, 4));
  m = fmaxf(m, shfl_xor_f(m, 8));
  const int q = (1 << (e.bits - 1)) - 1;
  int n = 0;
  uint32_t packed[EPL / 4];
#pragma unroll
  for (int w = 0; w < EPL / 4; ++w) packed[w] = 0u;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const int c = m > 0.f ? quant_elem<T>(v[k], m, q) : 0;
    n += c * c;
    packed[k / 4] |= ((uint32_t)c & 0xFFu) << (8 * (k % 4));
  }
  n += __shfl_xor(n, 1, FASTAR_WAVE);
  n += __shfl_xor(n, 2, FASTAR_WAVE);
  n += __shfl_xor(n, 4, FASTAR_WAVE);
  n += __shfl_xor(n, 8, FASTAR_WAVE);
  int8_t* crow = e.codes + r * D + sub * EPL;
  if (EPL == 8) *reinterpret_cast<uint2*>(crow) = make_uint2(packed[0], packed[EPL / 4 - 1]);
  else *reinterpret_cast<uint32_t*>(crow) = packed[0];
  if (sub == 0) {
    e.norm2[r] = n;
    if (e.rn) e.rn[r] = n > 0 ? (float)(1.0 / sqrt((double)n)) : 0.f;
    if (e.bias) e.bias[r] = valid ? 0.f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// exact comparisons on integer codes
// ---------------------------------------------------------------------------
// cos_a > cos_b for cosines d / sqrt(n * c) sharing the factor c (a zero
// norm means cosine 0)
__device__ __forceinline__ bool cos_greater(int da, int na, int db, int nb) {
  if (na == 0) da = 0;
  if (nb == 0) db = 0;
  const int sa = (da > 0) - (da < 0), sb = (db > 0) - (db < 0);
  if (sa != sb) return sa > sb;
  if (sa == 0) return false;
  const uint64_t l = (uint64_t)((int64_t)da * da) * (uint64_t)nb;
  const uint64_t r = (uint64_t)((int64_t)db * db) * (uint64_t)na;
  return sa > 0 ? l > r : l < r;
}

// tau as tm 2^-k (tm odd, or k = 0), sign ts
struct Tau {
  float f;
  uint32_t tm;
  int k, ts;
};

// d / sqrt(nn) >= tau exactly (nn = 0: cosine 0)
__device__ __forceinline__ bool cos_at_least(int d, uint64_t nn, const Tau& t) {
  if (nn == 0) d = 0;
  if (t.f > 1.f) return false;
  if (t.f <= -1.f) return true;
  if (t.ts == 0) return d >= 0;
  if (t.ts > 0 && d <= 0) return false;
  if (t.ts < 0 && d >= 0) return true;
  // |d| / sqrt(nn) against |tau|: d^2 2^(2k) against tm^2 nn
  const uint64_t d2 = (uint64_t)((int64_t)d * d);
  const int bl = 64 - __builtin_clzll(d2);
  bool larger;  // d^2 > tau^2 nn
  bool equal = false;
  if (bl + 2 * t.k >= 127) {
    larger = true;  // tm^2 nn < 2^90
  } else {
    const unsigned __int128 L = (unsigned __int128)d2 << (2 * t.k);
    const unsigned __int128 R = (unsigned __int128)((uint64_t)t.tm * t.tm) * nn;
    larger = L > R;
    equal = L == R;
  }
  // tau > 0, d > 0: cos >= tau iff d^2 >= tau^2 nn;  tau < 0, d < 0: iff d^2 <= tau^2 nn
  return t.ts > 0 ? (larger || equal) : !larger;
}

// exact code dot product of two rows (D bytes, 16-byte aligned)
template <int D>
__device__ __forceinline__ int code_dot(const int8_t* a, const int8_t* b) {
  int s = 0;
#pragma unroll
  for (int w = 0; w < D / 16; ++w) {
    const int4 x = reinterpret_cast<const int4*>(a)[w];
    const int4 y = reinterpret_cast<const int4*>(b)[w];
    s = __builtin_amdgcn_sdot4(x.x, y.x, s, false);
    s = __builtin_amdgcn_sdot4(x.y, y.y, s, false);
    s = __builtin_amdgcn_sdot4(x.z, y.z, s, false);
    s = __builtin_amdgcn_sdot4(x.w, y.w, s, false);
  }
  return s;
}

// ---------------------------------------------------------------------------
// match
// ---------------------------------------------------------------------------
struct QMatchArgs {
  int H, T, F;
  int ntab, moff;  // tables per head; the matcher table of frame f is f + 1 + moff
  Tau tau;
  const int8_t* codes;
  const int32_t* norm2;
  const float* rn;
  const float* bias;
  int32_t* ptgt;
  int32_t* pdot;
  float* pcos;
  fastar_diag_t* diag;
};

// bounds: a float32 score d * rn (d exact, rn correctly rounded) is within
// 2^-23 relative of d / sqrt(n); its cosine estimate score * rn_key within
// 2^-22; decisions closer than these are redone exactly
constexpr float kArgRel = 0x1p-21f;
constexpr float kTauAbs = 0x1p-20f;

// running best / second best score and the best's index; equal scores keep
// the earlier (smaller) index, so the result does not depend on the order
// lanes merge in
struct QTop {
  float c1, c2;
  int best;
  __device__ __forceinline__ void merge(float oc1, float oc2, int ob) {
    const bool o = ob >= 0 && (oc1 > c1 || (oc1 == c1 && (uint32_t)ob < (uint32_t)best));
    const float lo = o ? c1 : oc1;
    const float w2 = o ? oc2 : c2;
    c2 = lo > w2 ? lo : w2;
    c1 = o ? oc1 : c1;
    best = o ? ob : best;
  }
};

// Candidates go through LDS in tiles of 64 shared by the workgroup's four
// waves (16-byte direct loads, double-buffered, each row's 16-byte pieces
// XOR-swizzled by the row so that the 8 rows one read touches hit distinct
// banks), with their 1 / norms and biases.
template <int D>
__global__ __launch_bounds__(256) void tcq_match_kernel(QMatchArgs a) {
  constexpr int KB = D / 64;          // 64-byte k-blocks of a row
  constexpr int kPieces = D / 16;     // 16-byte pieces of a row
  constexpr int kRowsPer = 64 / kPieces;  // rows one 64-lane 16-byte load fills
  constexpr int kLoadsPerWave = kPieces / 4;
  __shared__ __attribute__((aligned(16))) int8_t ctA[64 * D];
  __shared__ __attribute__((aligned(16))) int8_t ctB[64 * D];
  __shared__ __attribute__((aligned(16))) float rtA[64];
  __shared__ __attribute__((aligned(16))) float rtB[64];
  __shared__ __attribute__((aligned(16))) float btA[64];
  __shared__ __attribute__((aligned(16))) float btB[64];
  const int h = blockIdx.y, f = blockIdx.z;
  const int lane = lane_id(), col = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int k0 = blockIdx.x * 64 + wave * 16;
  const int T = a.T;
  // a wave past the last key still loads its share of the tiles
  const bool wact = k0 < T;
  const int64_t tk = ((int64_t)h * a.ntab + f + 1 + a.moff) * T;  // matcher table rows (keys or queries)
  const int64_t tc = ((int64_t)h * a.ntab + f) * T;                // candidate table rows
  const int8_t* kc = a.codes + tk * D;
  const int8_t* cc = a.codes + tc * D;
  const float* crn = a.rn + tc;
  const float* cbias = a.bias + tc;
  // B operand: key k0 + col, bytes 16 g .. + 16 of each k-block
  const int key = wact && k0 + col < T ? k0 + col : T - 1;
  v4i32_t kb[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) kb[b] = *reinterpret_cast<const v4i32_t*>(kc + (int64_t)key * D + 64 * b + 16 * g);
  // tile t's rows (row r's piece p at position p ^ (r % kPieces)), 1 / norms
  // and biases; rows past the end repeat the last (masked when scored)
  auto load_tile = [&](int t, int8_t* ct, float* rt, float* bt) {
    const int c0 = t * 64;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int blk = wave * kLoadsPerWave + i;
      const int row = blk * kRowsPer + lane / kPieces;
      const int pc = lane % kPieces;
      const int c = min(c0 + row, T - 1);
      __builtin_amdgcn_global_load_lds((const void*)(cc + (int64_t)c * D + 16 * (pc ^ (row % kPieces))),
                                       (__attribute__((address_space(3))) void*)(ct + blk * 1024), 16, 0, 0);
    }
    const int c = min(c0 + lane, T - 1);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((const void*)(crn + c), (__attribute__((address_space(3))) void*)rt, 4, 0,
                                       0);
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((const void*)(cbias + c), (__attribute__((address_space(3))) void*)bt, 4,
                                       0, 0);
  };
  // running top two of the lane's scores; best holds the candidate minus
  // 4 g (the lane's offset within a block) until the tiles are done
  QTop t{-INFINITY, -INFINITY, -1};
  // the wave's 16 keys against tile ti's candidates.  BIASED: the frontier
  // (f == 0) may hold candidates without a group (bias -inf); TAIL: the last
  // tile's rows past the end
  auto compute = [&](auto biased_c, auto tail_c, int ti, const int8_t* ct, const float* rt, const float* bt) {
    constexpr bool BIASED = decltype(biased_c)::value, TAIL = decltype(tail_c)::value;
    const int c0 = ti * 64;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (TAIL && c0 + 16 * cb >= T) break;
      const int row = 16 * cb + col;
      v4i32_t acc = {0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const v4i32_t ca = *reinterpret_cast<const v4i32_t*>(ct + row * D + 16 * ((4 * b + g) ^ (row % kPieces)));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca, kb[b], acc, 0, 0, 0);
      }
      // acc[i] = code dot of candidate c0 + 16 cb + 4 g + i with key k0 + col
      const float4 r4 = *reinterpret_cast<const float4*>(rt + 16 * cb + 4 * g);
      const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BIASED) {
        const float4 b4 = *reinterpret_cast<const float4*>(bt + 16 * cb + 4 * g);
        bv[0] = b4.x;
        bv[1] = b4.y;
        bv[2] = b4.z;
        bv[3] = b4.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cr = c0 + 16 * cb + i;  // the candidate less 4 g (uniform)
        float s = BIASED ? fmaf((float)acc[i], rv[i], bv[i]) : (float)acc[i] * rv[i];
        if (TAIL) s = cr + 4 * g < T ? s : -INFINITY;
        const float c1o = t.c1;
        t.c2 = __builtin_amdgcn_fmed3f(s, c1o, t.c2);
        t.best = s > c1o ? cr : t.best;
        t.c1 = __builtin_amdgcn_fmed3f(s, c1o, INFINITY);  // the larger (no NaN here)
      }
    }
  };
  using yes = std::true_type;
  using no = std::false_type;
  const int ntile = (T + 63) / 64;
  // tile t + 1 loads while tile t is scored; before the barrier each wave
  // waits for its own loads of tile t, after it every wave's have landed and
  // every wave is done with tile t - 1, whose buffers tile t + 1 takes
  auto step = [&](int ti, const int8_t* ct, const float* rt, const float* bt, int8_t* cn, float* rn2,
                  float* bn) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (ti + 1 < ntile) load_tile(ti + 1, cn, rn2, bn);
    if (!wact) return;
    const bool tail = ti * 64 + 64 > T;
    if (f == 0) {
      if (tail) compute(yes{}, yes{}, ti, ct, rt, bt);
      else compute(yes{}, no{}, ti, ct, rt, bt);
    } else {
      if (tail) compute(no{}, yes{}, ti, ct, rt, bt);
      else compute(no{}, no{}, ti, ct, rt, bt);
    }
  };
  load_tile(0, ctA, rtA, btA);
  for (int ti = 0; ti < ntile; ti += 2) {
    step(ti, ctA, rtA, btA, ctB, rtB, btB);
    if (ti + 1 < ntile) step(ti + 1, ctB, rtB, btB, ctA, rtA, btA);
  }
  if (!wact) return;  // the whole wave; no barrier follows
  if (t.best >= 0) t.best += 4 * g;
  // the four lanes of a key (l, l ^ 16, l ^ 32, l ^ 48)
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    const float oc1 = shfl_xor_f(t.c1, m), oc2 = shfl_xor_f(t.c2, m);
    const int ob = shfl_xor_i(t.best, m);
    t.merge(oc1, oc2, ob);
  }
  const bool own = lane < 16 && k0 + col < T;
  const int nkey = a.norm2[tk + key];
  const float rk = a.rn[tk + key];
  int prop = -1, dot = 0;
  float pc = 0.f;
  bool amb = false;
  if (own && t.best >= 0) {
    const float cb = t.c1 * rk;
    const bool arg_amb = t.c2 > -INFINITY && t.c1 - t.c2 <= kArgRel * fmaxf(fabsf(t.c1), fabsf(t.c2));
    if (cb < a.tau.f - kTauAbs) {
      prop = -1;  // certainly below tau
    } else if (cb >= a.tau.f + kTauAbs && !arg_amb) {
      prop = t.best;
      pc = cb;
    } else {
      amb = true;
    }
  }
  // keys the float32 bound cannot decide: the whole wave, exactly (counted
  // per wave and added to diag once)
  uint64_t ab = ballot64(amb);
  const unsigned nfb = (unsigned)__popcll(ab);
  while (ab) {
    const int src = __builtin_ctzll(ab);
    ab &= ab - 1;
    const int ks = __shfl(key, src, FASTAR_WAVE);
    const int ns = __shfl(nkey, src, FASTAR_WAVE);
    const int8_t* krow = kc + (int64_t)ks * D;
    int bd = 0, bn = 0, bi = -1;
    for (int i = lane; i < T; i += FASTAR_WAVE) {
      if (cbias[i] != 0.f) continue;  // no candidate
      const int di = code_dot<D>(krow, cc + (int64_t)i * D);
      const int ni = a.norm2[tc + i];
      if (bi < 0 || cos_greater(di, ni, bd, bn)) {
        bd = di;
        bn = ni;
        bi = i;
      }
    }
    // wave maximum, ties to the smaller index (each lane's best is its smallest-index maximum)
#pragma unroll
    for (int m = 1; m < FASTAR_WAVE; m <<= 1) {
      const int od = __shfl_xor(bd, m, FASTAR_WAVE), on = __shfl_xor(bn, m, FASTAR_WAVE);
      const int oi = __shfl_xor(bi, m, FASTAR_WAVE);
      const bool take = oi >= 0 && (bi < 0 || cos_greater(od, on, bd, bn) ||
                                    (!cos_greater(bd, bn, od, on) && oi < bi));
      if (take) {
        bd = od;
        bn = on;
        bi = oi;
      }
    }
    if (lane == src) {
      const bool ok = bi >= 0 && cos_at_least(bd, (uint64_t)ns * (uint64_t)bn, a.tau);
      prop = ok ? bi : -1;
      dot = bd;
      pc = (bn > 0 && ns > 0) ? (float)((double)bd / sqrt((double)ns * (double)bn)) : 0.f;
    }
  }
  if (a.diag && lane == 0 && nfb) atomicAdd(&a.diag->merge_fallbacks, nfb);
  if (own) {
    if (prop >= 0 && !amb) dot = code_dot<D>(kc + (int64_t)key * D, cc + (int64_t)prop * D);
    const int64_t o = ((int64_t)h * a.F + f) * T + key;
    a.ptgt[o] = prop;
    a.pdot[o] = dot;
    a.pcos[o] = pc;
  }
}

// ---------------------------------------------------------------------------
// resolution
// ---------------------------------------------------------------------------
struct QResolveArgs {
  int H, T, F;
  int ntab, moff;
  const int32_t* norm2;     // key norms: tables 1..F
  const int32_t* ptgt;
  const int32_t* pdot;
  const float* pcos;
  const int32_t* frontier;  // [H][T]
  int32_t* link;
  int32_t* nextj;
  int32_t* ocnt;
  int nblk;
};

// one workgroup of 1024 threads per (frame, head); T <= 2048
constexpr int kResThreads = 1024;
constexpr int kResPer = 2;

__global__ __launch_bounds__(kResThreads) void tcq_resolve_kernel(QResolveArgs a) {
  __shared__ int32_t start[2048 + 1];
  __shared__ int32_t list[2048];
  __shared__ int32_t wsum[kResThreads / FASTAR_WAVE];
  const int f = blockIdx.x, h = blockIdx.y, T = a.T;
  const int64_t po = ((int64_t)h * a.F + f) * T;
  const int64_t kn = ((int64_t)h * a.ntab + f + 1 + a.moff) * T;
  int tg[kResPer], dj[kResPer], nj[kResPer];
  float cj[kResPer];
#pragma unroll
  for (int u = 0; u < kResPer; ++u) {
    const int j = threadIdx.x + u * kResThreads;
    const bool v = j < T;
    tg[u] = v ? a.ptgt[po + j] : -1;
    dj[u] = v ? a.pdot[po + j] : 0;
    cj[u] = v ? a.pcos[po + j] : 0.f;
    nj[u] = v ? a.norm2[kn + j] : 0;
  }
  for (int i = threadIdx.x; i <= T; i += kResThreads) start[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kResPer; ++u)
    if (tg[u] >= 0) atomicAdd(&start[tg[u]], 1);
  __syncthreads();
  // exclusive scan of the T counts (two per thread)
  {
    const int i0 = 2 * threadIdx.x;
    const int c0 = i0 < T ? start[i0] : 0, c1 = i0 + 1 < T ? start[i0 + 1] : 0;
    const int loc = c0 + c1;
    const int incl = (int)wave_incl_scan_dpp((uint32_t)loc);
    const int w = threadIdx.x >> 6;
    if (lane_id() == FASTAR_WAVE - 1) wsum[w] = incl;
    __syncthreads();
    const int lw = lane_id() < kResThreads / FASTAR_WAVE ? wsum[lane_id()] : 0;
    const int base = incl - loc + wave_sum_dpp(lane_id() < w ? lw : 0);
    __syncthreads();
    if (i0 < T) start[i0] = base;
    if (i0 + 1 < T) start[i0 + 1] = base + c0;
    if (threadIdx.x == kResThreads - 1) start[T] = base + loc;
  }
  __syncthreads();
  // scatter the proposers by candidate (order within a candidate does not matter)
  __shared__ int32_t cur[2048];
  for (int i = threadIdx.x; i < T; i += kResThreads) cur[i] = start[i];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kResPer; ++u)
    if (tg[u] >= 0) list[atomicAdd(&cur[tg[u]], 1)] = threadIdx.x + u * kResThreads;
  __syncthreads();
  const int32_t* fr = a.frontier + (int64_t)h * T;
#pragma unroll
  for (int u = 0; u < kResPer; ++u) {
    const int j = threadIdx.x + u * kResThreads;
    if (j >= T) continue;
    bool win = tg[u] >= 0;
    if (win) {
      // beaten by another proposer of the candidate with a larger cosine, or an equal one and a smaller index
      for (int p = start[tg[u]]; p < start[tg[u] + 1]; ++p) {
        const int j2 = list[p];
        if (j2 == j) continue;
        const float c2 = a.pcos[po + j2];
        bool beats;
        if (fabsf(c2 - cj[u]) > kTauAbs) {
          beats = c2 > cj[u];
        } else {
          const int d2 = a.pdot[po + j2], n2 = a.norm2[kn + j2];
          beats = cos_greater(d2, n2, dj[u], nj[u]) || (!cos_greater(dj[u], nj[u], d2, n2) && j2 < j);
        }
        if (beats) {
          win = false;
          break;
        }
      }
    }
    int lk = -1;
    if (win) {
      lk = f == 0 ? fr[tg[u]] : tg[u];
      if (f > 0) a.nextj[((int64_t)h * a.F + f - 1) * T + tg[u]] = j;
    }
    a.link[po + j] = lk;
    if (lk < 0) atomicAdd(&a.ocnt[(int64_t)h * (a.nblk + 1) + ((f * T + j) >> 6)], 1);
  }
}

template <typename T, int D>
hipError_t merge_quant_td(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                          const fastar_tensor_t* qn, const int32_t* kb, int F, float tau, int bits,
                          int32_t* group_of_new,
                          int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws, const QuantWs& q,
                          fastar_diag_t* diag, hipStream_t s) {
  const int H = c.heads, Tf = c.tokens_per_frame;
  MergeArgs m{};
  m.H = H;
  m.Tf = Tf;
  m.cap = c.capacity;
  m.F = F;
  m.nbits = c.n_bits;
  m.kb_stride = ws.kb_stride > 0 ? ws.kb_stride : (int64_t)F * Tf;
  m.link = ws.link;
  m.ocnt = ws.ocnt;
  m.nextj = ws.nextj;
  const int nblk = ocnt_blocks(m);
  EncArgs e{};
  e.mode = 1;
  e.H = H;
  e.bits = bits;
  e.x = kn.data;
  e.sh = kn.stride_head;
  e.st = kn.stride_token;
  e.rep_k = c.rep_k;
  e.frontier = c.frontier;
  e.n_groups = c.n_groups;
  e.T = Tf;
  e.F = F;
  e.cap = c.capacity;
  e.nextj = ws.nextj;
  e.ocnt = ws.ocnt;
  e.nblk = nblk;
  e.codes = q.codes;
  e.norm2 = q.norm2;
  e.rn = q.rn;
  e.bias = q.bias;
  e.qd = qn != nullptr;
  if (qn) {
    e.q = qn->data;
    e.qsh = qn->stride_head;
    e.qst = qn->stride_token;
  }
  const int ntab = F + 1 + (qn ? F : 0);
  hipLaunchKernelGGL((tcq_encode_kernel<T, D>), dim3((unsigned)((Tf + 15) / 16), (unsigned)ntab, (unsigned)H),
                     dim3(256), 0, s, e);
  QMatchArgs ma{};
  ma.H = H;
  ma.T = Tf;
  ma.F = F;
  ma.ntab = ntab;
  ma.moff = qn ? F : 0;
  {
    Tau t;
    t.f = tau;
    t.ts = (tau > 0.f) - (tau < 0.f);
    int ex = 0;
    const double fr = frexp(fabs((double)tau), &ex);  // |tau| = fr 2^ex, fr in [0.5, 1)
    uint64_t mant = (uint64_t)ldexp(fr, 24);          // exact: 24 significant bits
    int k = 24 - ex;
    while (mant && (mant & 1) == 0 && k > 0) {
      mant >>= 1;
      --k;
    }
    t.tm = (uint32_t)mant;
    t.k = k;
    ma.tau = t;
  }
  ma.codes = q.codes;
  ma.norm2 = q.norm2;
  ma.rn = q.rn;
  ma.bias = q.bias;
  ma.ptgt = q.ptgt;
  ma.pdot = q.pdot;
  ma.pcos = q.pcos;
  ma.diag = diag;
  hipLaunchKernelGGL((tcq_match_kernel<D>), dim3((unsigned)((Tf + 63) / 64), (unsigned)H, (unsigned)F), dim3(256),
                     0, s, ma);
  QResolveArgs ra{};
  ra.H = H;
  ra.T = Tf;
  ra.F = F;
  ra.ntab = ntab;
  ra.moff = qn ? F : 0;
  ra.norm2 = q.norm2;
  ra.ptgt = q.ptgt;
  ra.pdot = q.pdot;
  ra.pcos = q.pcos;
  ra.frontier = c.frontier;
  ra.link = ws.link;
  ra.nextj = ws.nextj;
  ra.ocnt = ws.ocnt;
  ra.nblk = nblk;
  hipLaunchKernelGGL(tcq_resolve_kernel, dim3((unsigned)F, (unsigned)H), dim3(kResThreads), 0, s, ra);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_merge_apply(c, kn, vn, kb, m, group_of_new, rep_offsets, rep_perm, ws, diag, s);
}

}  // namespace

size_t quant_workspace_bytes(int heads, int T, int F, int dim, bool query_driven) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)heads * (F + 1 + (query_driven ? F : 0)) * T, props = (size_t)heads * F * T;
  return al(rows * dim) + 3 * al(4 * rows) + 3 * al(4 * props);
}

QuantWs quant_carve(int heads, int T, int F, int dim, bool query_driven, void* ws) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)heads * (F + 1 + (query_driven ? F : 0)) * T, props = (size_t)heads * F * T;
  char* w = (char*)ws;
  QuantWs q;
  q.codes = (int8_t*)w;
  w += al(rows * dim);
  q.norm2 = (int32_t*)w;
  w += al(4 * rows);
  q.rn = (float*)w;
  w += al(4 * rows);
  q.bias = (float*)w;
  w += al(4 * rows);
  q.ptgt = (int32_t*)w;
  w += al(4 * props);
  q.pdot = (int32_t*)w;
  w += al(4 * props);
  q.pcos = (float*)w;
  return q;
}

hipError_t launch_scalar_codes(const fastar_tensor_t& x, int bits, int8_t* codes, int32_t* norm2,
                               hipStream_t s) {
  const int64_t rows = (int64_t)x.heads * x.tokens;
  if (rows == 0) return hipSuccess;
  EncArgs e{};
  e.mode = 0;
  e.H = x.heads;
  e.bits = bits;
  e.x = x.data;
  e.sh = x.stride_head;
  e.st = x.stride_token;
  e.N = x.tokens;
  e.codes = codes;
  e.norm2 = norm2;
  const dim3 grid((unsigned)((x.tokens + 15) / 16), 1u, (unsigned)x.heads), block(256);
  if (x.dtype == FASTAR_BF16) {
    if (x.dim == 64) hipLaunchKernelGGL((tcq_encode_kernel<uint16_t, 64>), grid, block, 0, s, e);
    else hipLaunchKernelGGL((tcq_encode_kernel<uint16_t, 128>), grid, block, 0, s, e);
  } else {
    if (x.dim == 64) hipLaunchKernelGGL((tcq_encode_kernel<float, 64>), grid, block, 0, s, e);
    else hipLaunchKernelGGL((tcq_encode_kernel<float, 128>), grid, block, 0, s, e);
  }
  return hipGetLastError();
}

hipError_t launch_tempcache_merge_quant(const fastar_cache_t& c, const fastar_tensor_t& k_new,
                                        const fastar_tensor_t& v_new, const fastar_tensor_t* q_new,
                                        const int32_t* k_new_bucket, int n_frames, float tau, int bits,
                                        int32_t* group_of_new, int32_t* rep_offsets, int32_t* rep_perm,
                                        const MergeWs& ws, const QuantWs& qws, fastar_diag_t* diag,
                                        hipStream_t s) {
  if (c.heads == 0 || n_frames == 0) return hipSuccess;
  if (c.dtype == FASTAR_BF16)
    return c.dim == 64 ? merge_quant_td<uint16_t, 64>(c, k_new, v_new, q_new, k_new_bucket, n_frames, tau, bits,
                                                      group_of_new, rep_offsets, rep_perm, ws, qws, diag, s)
                       : merge_quant_td<uint16_t, 128>(c, k_new, v_new, q_new, k_new_bucket, n_frames, tau, bits,
                                                       group_of_new, rep_offsets, rep_perm, ws, qws, diag, s);
  return c.dim == 64 ? merge_quant_td<float, 64>(c, k_new, v_new, q_new, k_new_bucket, n_frames, tau, bits,
                                                 group_of_new, rep_offsets, rep_perm, ws, qws, diag, s)
                     : merge_quant_td<float, 128>(c, k_new, v_new, q_new, k_new_bucket, n_frames, tau, bits,
                                                  group_of_new, rep_offsets, rep_perm, ws, qws, diag, s);
}

}  // namespace fastar
