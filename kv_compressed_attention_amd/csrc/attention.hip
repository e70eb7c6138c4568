// Bucket-restricted flash attention (AnnSA / AnnCA) on gfx950.
//
// o_q = sum_j softmax_j(scale * q.k_j + bias_j) v_j, where the key set of q
// is the keys of its bucket(s) (AnnSA: paperlayer.ai section 5 "AnnSA",
// gist.science AnnSA), a kept-prompt list (AnnCA), or all keys; bias_j is
// ln m_j for a TempCache group of m_j merged keys (Lemma 5.1, paperlayer.ai
// appendix A).
//
// bf16 kernel layout.  A wave owns 16 query rows, taken in index (bucket)
// order, so a wave's rows usually share one or a few buckets.  It walks the
// distinct buckets of its rows (both probes) in ascending order; for each it
// streams that bucket's keys in chunks of 32 with rows outside the bucket
// masked.  Per chunk:
//   S^T[32 keys x 16 rows] = K Q^T   two v_mfma_f32_16x16x32_bf16 groups,
//                                      K gathered straight from HBM (each lane
//                                      reads 64 contiguous bytes of one key);
//   online softmax in float32 with exp2, row max shared by the 4 lanes of a row;
//   O^T[d x 16 rows] += V^T P^T         d/16 MFMAs.  P^T comes out of S^T's
//                                      accumulator layout with no shuffles; V^T
//                                      is built in registers: each lane loads 16
//                                      contiguous bytes of 8 keys and transposes
//                                      8x8 16-bit values, so V needs no LDS.
// The dims of O^T are interleaved (row r of block b is dim (d/16) r + b) so
// that every lane finally holds 32 (d=128) contiguous output dims.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate: vector memory count 0, the other counters unconstrained
constexpr int kWaitVm0 = 0x0F70;
constexpr float kLn2 = 0.6931471805599453f;

template <int NB>
struct VRow;
template <>
struct VRow<8> {  // d = 128: 8 bf16 per lane per key
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  // the 32-bit word holding dim b (its half: b & 1)
  __device__ __forceinline__ uint32_t word(int b) const {
    return (b < 2) ? u.x : (b < 4) ? u.y : (b < 6) ? u.z : u.w;
  }
};
template <>
struct VRow<4> {  // d = 64: 4 bf16 per lane per key
  uint2 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ uint32_t word(int b) const { return (b < 2) ? u.x : u.y; }
};


// MODE: 0 bucket, 1 key list, 2 dense.  Every head's k and v rows lie within
// 4 GiB of the head's first row (checked by the caller), so row offsets are
// 32-bit byte offsets from the head's base.
template <int D, int P, int MODE>
__global__ __launch_bounds__(256, 4) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t q_sh, int64_t q_st, int64_t Nq,
    const int32_t* __restrict__ q_bucket, const int32_t* __restrict__ q_perm,
    const uint16_t* __restrict__ k, int64_t k_sh, int64_t k_st,
    const uint16_t* __restrict__ v, int64_t v_sh, int64_t v_st, int64_t Nk,
    const float* __restrict__ key_bias, const int32_t* __restrict__ k_offsets,
    const int32_t* __restrict__ k_perm, int nbits, const int32_t* __restrict__ key_list,
    const int32_t* __restrict__ n_key_list, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int H) {
  constexpr int NC = D / 32;  // k-chunks of the QK^T contraction
  constexpr int NB = D / 16;  // 16-dim output blocks
  // rows of the V chunk one 16-byte-per-lane LDS load fills
  constexpr int kVRows = 64 * 16 / (2 * D);
  __shared__ __attribute__((aligned(16))) uint16_t vlds[4][32 * D];
  __shared__ __attribute__((aligned(16))) float blds[4][32];
  // logical block (row block, head), XCD-grouped
  const int64_t nbx = (Nq + 63) / 64;
  const int64_t lb = xcd_block(blockIdx.x, nbx * H);
  if (lb >= nbx * H) return;
  const int h = (int)(lb / nbx);
  const int64_t bx = lb - (int64_t)h * nbx;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  uint16_t* vbuf = vlds[wave];
  float* bbuf = blds[wave];
  const int64_t r0 = bx * 64 + wave * 16;
  if (r0 >= Nq) return;
  const int64_t r = r0 + col;
  const bool rvalid = r < Nq;
  int64_t t = r0;
  if (rvalid) t = (MODE == 0) ? (int64_t)q_perm[(int64_t)h * Nq + r] : r;

  // B operand of S^T = K Q^T: query row `col`, dims 32c + 8g .. +8
  bf16x8_t qop[NC];
  {
    const uint16_t* qrow = q + (int64_t)h * q_sh + t * q_st;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      if (!rvalid) u = make_uint4(0u, 0u, 0u, 0u);
      qop[c] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  float m = -INFINITY;
  float lsum = 0.f;
  f32x4_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const char* kh = reinterpret_cast<const char*>(k + (int64_t)h * k_sh);
  const char* vh = reinterpret_cast<const char*>(v + (int64_t)h * v_sh);
  const uint32_t kst_b = (uint32_t)(k_st * 2), vst_b = (uint32_t)(v_st * 2);
  const float* bh = key_bias ? key_bias + (int64_t)h * Nk : nullptr;
  const int32_t* idx_h = nullptr;
  if (MODE == 0) idx_h = k_perm + (int64_t)h * Nk;
  if (MODE == 1) idx_h = key_list + (int64_t)h * Nk;

  // passes: the distinct buckets of the wave's rows in ascending order (MODE
  // 0; lane i holds pass i's bucket and key range), or one pass over the list
  // or all keys.  Every pass's key range is loaded at once.  pr0 / pr1: the
  // passes of this row's buckets.
  int b0 = INT_MAX, b1 = INT_MAX;
  if (MODE == 0 && rvalid) {
    const int32_t* qb = q_bucket + ((int64_t)h * Nq + t) * P;
    b0 = qb[0];
    if (P == 2) b1 = qb[1];
  }
  int npass = 0, xs = INT_MAX, pkb = 0, pke = 0, pr0 = -1, pr1 = -1;
  if (MODE == 0) {
    int c0 = b0, c1 = b1;
    while (true) {
      const int X = wave_min_dpp(min(c0, c1));
      if (X == INT_MAX) break;
      if (l == npass) xs = X;
      if (c0 == X) {
        c0 = INT_MAX;
        pr0 = npass;
      }
      if (c1 == X) {
        c1 = INT_MAX;
        pr1 = npass;
      }
      ++npass;
    }
    if (l < npass) {
      const int32_t* off = k_offsets + (int64_t)h * ((1 << nbits) + 1) + xs;
      pkb = off[0];
      pke = off[1];
    }
  } else {
    npass = 1;
    int64_t ke = Nk;
    if (MODE == 1) {
      const int64_t nl = n_key_list[h];
      ke = nl < 0 ? 0 : (nl < Nk ? nl : Nk);
    }
    pke = (int)ke;
    if (rvalid) pr0 = 0;
  }
  // the passes' key ranges, concatenated: pass p's keys are slots
  // pre_p .. pre_p + len_p - 1 of the wave's key list
  const int len = l < npass ? pke - pkb : 0;
  // lane p < npass: pre = slots of the passes before p; the rows' slot
  // ranges, [lo0, lo0 + n0) and, with two probes, [lo1, lo1 + n1), from the
  // same walk over the (few) passes with wave-uniform reads
  int pre = 0, total = 0;
  uint32_t lo0 = 0u, n0 = 0u, lo1 = 0u, n1 = 0u;
  for (int p = 0; p < npass; ++p) {
    const int lp = __builtin_amdgcn_readlane(len, p);
    if (l == p) pre = total;
    if (pr0 == p) {
      lo0 = (uint32_t)total;
      n0 = (uint32_t)lp;
    }
    if (P == 2 && pr1 == p) {
      lo1 = (uint32_t)total;
      n1 = (uint32_t)lp;
    }
    total += lp;
  }
  // key of list slot j (past the end: the last slot's, which no row uses);
  // the pass is found with wave-uniform reads of the pass table
  const int kb_pre = pkb - pre;  // slot j of pass p is position j + kb_pre_p
  auto slot_key = [&](int j) {
    const int jc = min(j, total - 1);
    int base = __builtin_amdgcn_readfirstlane(kb_pre);
    for (int q2 = 1; q2 < npass; ++q2) {
      const int pq = __builtin_amdgcn_readlane(pre, q2);
      const int bq = __builtin_amdgcn_readlane(kb_pre, q2);
      base = pq <= jc ? bq : base;
    }
    const int kk = jc + base;
    return (MODE == 2) ? kk : idx_h[kk];
  };
  // Chunks of 32 list slots: at chunk kc lane j < 32 holds the key of
  // chunk slot j in ks, and the next chunk's keys load during the chunk.
  int ks = total > 0 ? slot_key(l) : 0;
  for (int kc = 0; kc < total; kc += 32) {
    const int ks_next = slot_key(kc + 32 + l);
    const uint32_t koff_l = (uint32_t)ks * kst_b;
    const uint32_t voff_l = (uint32_t)ks * vst_b;
    // the chunk's 32 V rows go straight to the wave's LDS buffer (slot j of
    // the chunk at row j), issued with the K gathers; V does not depend on
    // the scores, and no registers hold it until the PV product
    // (all row offsets are fetched from their lanes before the first load)
    uint32_t vo[32 / kVRows];
#pragma unroll
    for (int i = 0; i < 32 / kVRows; ++i)
      vo[i] = (uint32_t)__shfl((int)voff_l, kVRows * i + l / (64 / kVRows), FASTAR_WAVE);
    uint32_t ko[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) ko[hf] = (uint32_t)__shfl((int)koff_l, 16 * hf + col, FASTAR_WAVE);
#pragma unroll
    for (int i = 0; i < 32 / kVRows; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(vh + (uint32_t)(vo[i] + (l % (64 / kVRows)) * 16)),
          (__attribute__((address_space(3))) void*)(vbuf + kVRows * i * D), 16, 0, 0);
    // the 32 biases: lane j < 32 loads chunk slot j's to bbuf[j]
    if (bh && l < 32)
      __builtin_amdgcn_global_load_lds((const void*)(bh + ks),
                                       (__attribute__((address_space(3))) void*)bbuf, 4, 0, 0);
    // K rows: lane (col, g) reads slot 16 hf + col, dims 32c + 8g .. +8
    uint4 kraw[2][NC];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const char* krow = kh + (uint32_t)(ko[hf] + 16u * g);
#pragma unroll
      for (int c = 0; c < NC; ++c) kraw[hf][c] = *reinterpret_cast<const uint4*>(krow + 64 * c);
    }
    // the MFMAs below wait for the K rows, which were issued after the V rows
    // and biases: every row load of the chunk has landed after this wait
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __asm__ volatile("" ::: "memory");
    float s[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // slot 4 hf + i <-> chunk row 16 hf + 4 g + i
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if (bh) {
        const float4 b4 = *reinterpret_cast<const float4*>(bbuf + 16 * hf + 4 * g);
        bias[0] = b4.x * kLog2e;
        bias[1] = b4.y * kLog2e;
        bias[2] = b4.z * kLog2e;
        bias[3] = b4.w * kLog2e;
      }
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kraw[hf][c]), qop[c], sacc, 0, 0, 0);
      // sacc[i] = score(list slot kc + 16 hf + 4 g + i, row col)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t j = (uint32_t)(kc + 16 * hf + 4 * g + i);
        bool in = j - lo0 < n0;
        if (P == 2) in = in || j - lo1 < n1;
        s[4 * hf + i] = in ? sacc[i] * scale_log2 + bias[i] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = max_xor32(max_xor16(mx));
    const float mnew = fmaxf(m, mx);
    const float base = (mnew == -INFINITY) ? 0.f : mnew;
    uint32_t pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(s[2 * i] - base), __builtin_amdgcn_exp2f(s[2 * i + 1] - base));
    // the sum of the rounded weights that the PV product uses
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                              __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
    // rescale the running sums only where a row's (finite) max went up
    if (ballot64(m != -INFINITY && mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - base);
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b][0] *= alpha;
        acc[b][1] *= alpha;
        acc[b][2] *= alpha;
        acc[b][3] *= alpha;
      }
    }
    lsum += psum;
    m = mnew;
    const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    // V^T operand: lane (dim-row col, group g), slot si <-> chunk row
    // 16 (si >> 2) + 4g + (si & 3), dims NB*col .. NB*col + NB - 1 (one per
    // output block), read back from LDS
    VRow<NB> vr[8];
#pragma unroll
    for (int si = 0; si < 8; ++si) vr[si].load(vbuf + (16 * (si >> 2) + 4 * g + (si & 3)) * D + NB * col);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // (slot 2i's dim, slot 2i+1's dim) in one byte permute per dword
      const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
      const uint4 w = make_uint4(__builtin_amdgcn_perm(vr[1].word(b), vr[0].word(b), sel),
                                 __builtin_amdgcn_perm(vr[3].word(b), vr[2].word(b), sel),
                                 __builtin_amdgcn_perm(vr[5].word(b), vr[4].word(b), sel),
                                 __builtin_amdgcn_perm(vr[7].word(b), vr[6].word(b), sel));
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w), pop, acc[b], 0, 0, 0);
    }
    ks = ks_next;
  }
  lsum = sum_xor32(sum_xor16(lsum));
  if (!rvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  // acc[b][i] = O[row col][NB*(4g+i) + b]: dims 4*NB*g .. 4*NB*g + 4*NB - 1
  uint32_t ow[2 * NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < NB; b += 2) ow[(i * NB + b) / 2] = pack_bf16x2(acc[b][i] * inv, acc[b + 1][i] * inv);
  uint16_t* orow = out + ((int64_t)h * Nq + t) * D + 4 * NB * g;
#pragma unroll
  for (int j = 0; j < NB / 2; ++j)
    reinterpret_cast<uint4*>(orow)[j] = make_uint4(ow[4 * j], ow[4 * j + 1], ow[4 * j + 2], ow[4 * j + 3]);
  if (lse && g == 0) lse[(int64_t)h * Nq + t] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
}

// fp32: one query row per lane on the vector ALUs (no fp32 MFMA rounding
// concerns; the fp32 workloads are small).
template <int D, int P, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, int64_t q_sh, int64_t q_st, int64_t Nq,
    const int32_t* __restrict__ q_bucket, const int32_t* __restrict__ q_perm,
    const float* __restrict__ k, int64_t k_sh, int64_t k_st, const float* __restrict__ v,
    int64_t v_sh, int64_t v_st, int64_t Nk, const float* __restrict__ key_bias,
    const int32_t* __restrict__ k_offsets, const int32_t* __restrict__ k_perm, int nbits,
    const int32_t* __restrict__ key_list, const int32_t* __restrict__ n_key_list, float scale,
    float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= Nq) return;
  const int64_t t = (MODE == 0) ? (int64_t)q_perm[(int64_t)h * Nq + r] : r;
  float qr[D], acc[D];
  const float* qrow = q + (int64_t)h * q_sh + t * q_st;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qrow[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, lsum = 0.f;
  const float* kh = k + (int64_t)h * k_sh;
  const float* vh = v + (int64_t)h * v_sh;
  const float* bh = key_bias ? key_bias + (int64_t)h * Nk : nullptr;
  int buckets[2] = {0, -1};
  int nseg = 1;
  if (MODE == 0) {
    const int32_t* qb = q_bucket + ((int64_t)h * Nq + t) * P;
    buckets[0] = qb[0];
    if (P == 2) {
      buckets[1] = qb[1];
      nseg = 2;
    }
  }
  for (int sgi = 0; sgi < nseg; ++sgi) {
    int64_t kbeg = 0, kend = Nk;
    const int32_t* idx = nullptr;
    if (MODE == 0) {
      const int32_t* off = k_offsets + (int64_t)h * ((1 << nbits) + 1) + buckets[sgi];
      kbeg = off[0];
      kend = off[1];
      idx = k_perm + (int64_t)h * Nk;
    } else if (MODE == 1) {
      const int64_t nl = n_key_list[h];
      kend = nl < 0 ? 0 : (nl < Nk ? nl : Nk);
      idx = key_list + (int64_t)h * Nk;
    }
    for (int64_t kk = kbeg; kk < kend; ++kk) {
      const int64_t key = idx ? idx[kk] : kk;
      const float* krow = kh + key * k_st;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], krow[d], s);
      s = s * scale + (bh ? bh[key] : 0.f);
      const float mnew = fmaxf(m, s);
      const float alpha = expf(m - mnew);
      const float p = expf(s - mnew);
      m = mnew;
      lsum = lsum * alpha + p;
      const float* vrow = vh + key * v_st;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vrow[d], acc[d] * alpha);
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* orow = out + ((int64_t)h * Nq + t) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  if (lse) lse[(int64_t)h * Nq + t] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
}

template <int D, int P, int MODE>
hipError_t launch3(const AttnArgs& a, hipStream_t s) {
  if (a.dtype == FASTAR_BF16) {
    const int64_t nb = (a.nq + 63) / 64 * a.heads;
    dim3 grid((unsigned)(FASTAR_XCDS * xcd_span(nb)));
    hipLaunchKernelGGL((attn_bf16_kernel<D, P, MODE>), grid, dim3(256), 0, s,
                       (const uint16_t*)a.q, a.q_sh, a.q_st, a.nq, a.q_bucket, a.q_perm,
                       (const uint16_t*)a.k, a.k_sh, a.k_st, (const uint16_t*)a.v, a.v_sh, a.v_st,
                       a.nk, a.key_bias, a.k_offsets, a.k_perm, a.n_bits, a.key_list,
                       a.n_key_list, a.scale * kLog2e, (uint16_t*)a.out, a.lse, a.heads);
  } else {
    dim3 grid((unsigned)((a.nq + 63) / 64), (unsigned)a.heads);
    hipLaunchKernelGGL((attn_f32_kernel<D, P, MODE>), grid, dim3(64), 0, s,
                       (const float*)a.q, a.q_sh, a.q_st, a.nq, a.q_bucket, a.q_perm,
                       (const float*)a.k, a.k_sh, a.k_st, (const float*)a.v, a.v_sh, a.v_st,
                       a.nk, a.key_bias, a.k_offsets, a.k_perm, a.n_bits, a.key_list,
                       a.n_key_list, a.scale, (float*)a.out, a.lse);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.mode == 0) return a.n_probes == 2 ? launch3<D, 2, 0>(a, s) : launch3<D, 1, 0>(a, s);
  if (a.mode == 1) return launch3<D, 1, 1>(a, s);
  return launch3<D, 1, 2>(a, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.heads == 0 || a.nq == 0) return hipSuccess;
  return a.dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace fastar
